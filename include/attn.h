/*
 * attn.h -- C ABI of the exact scaled-dot-product attention forward library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (defined on the pages "AI 大模型之 FlashAttention_02", sections 3.1 and
 * 4.1, and "Inside FlashAttention-3", section 2) is, for every batch b and head h,
 *
 *     S   = scale * Q K^T                      (Sq x Sk, never stored)
 *     S_ij = -inf where key j is masked
 *     O   = softmax(S) V,   lse_i = ln sum_j exp(S_ij)
 *
 * computed tile by tile with the two-level online softmax (running row maximum m,
 * running sum l, rescale factor exp(m_old - m_new), division by l deferred to the
 * write-back), so that the score matrix never reaches device memory.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  Layout     Q is [B, H, Sq, d]; K and V are [B, H, Sk, d]; O is [B, H, Sq, d] fp32;
 *             lse is [B, H, Sq] fp32.  All contiguous, row-major, in device memory.
 *  Types      ATTN_F32: float; ATTN_BF16: bfloat16 bit patterns (uint16);
 *             ATTN_FP8_E4M3: OCP FP8 E4M3FN codes (uint8, bias 7, max 448, no inf).
 *  Alignment  every pointer must be 16-byte aligned.
 *  Head dim   d must be 64, 128 or 256.  Anything else is refused (no fallback).
 *  Masks      causal = 0: none.  causal = 1: key j is hidden from query i when
 *             j > i + (Sk - Sq) (aligned to the bottom-right corner; the usual j > i
 *             when Sq == Sk).  A query row that sees no key gets O = 0, lse = -inf.
 *  scale      applied as the given fp32 value; must be finite and > 0.
 *  lse        natural log of the sum of exp of the row's visible scaled scores.
 *  Streams    `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *             asynchronous on that stream; results are valid once the stream has
 *             reached that point.  The library never allocates, frees or
 *             synchronises; the caller owns every buffer and keeps it alive until
 *             the stream is done with it.  Calls are thread-safe.
 *  Errors     every call returns an attn_status.  All arguments are checked before
 *             anything is launched, so a refused call leaves every output untouched.
 *             A failed launch returns ATTN_ERR_HIP and records the HIP error code,
 *             readable with attn_last_hip_error() on the calling thread.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_F32 = 0,
  ATTN_BF16 = 1,
  ATTN_FP8_E4M3 = 2
} attn_dtype;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,        /* a required pointer is NULL                              */
  ATTN_ERR_SHAPE = 2,       /* B, H, Sq or Sk < 1, or sizes too large to index         */
  ATTN_ERR_ALIGN = 3,       /* a pointer is not 16-byte aligned                         */
  ATTN_ERR_UNSUPPORTED = 4, /* head dim or dtype not supported                          */
  ATTN_ERR_WORKSPACE = 5,   /* split-KV workspace smaller than attn_splitkv_workspace_bytes */
  ATTN_ERR_HIP = 6,         /* the kernel launch failed (see attn_last_hip_error)      */
  ATTN_ERR_ARG = 7          /* causal not 0/1, scale or a descale not finite and > 0,
                               num_splits out of [1, ATTN_MAX_SPLITS]                  */
} attn_status;

#define ATTN_MAX_SPLITS 4096

/*
 * attn_fwd -- fused attention forward: O and lse for every (b, h, query row).
 *
 * One workgroup per (b, h, tile of query rows) sweeps all visible keys (the
 * sequence-level work partition of "AI 大模型之 FlashAttention_02", section "From
 * head-level to sequence-level parallelism"); no workgroup ever reduces with another.
 * For ATTN_FP8_E4M3 the codes are used as they are: fold any q/k descale into
 * `scale` and multiply O by the v descale afterwards (attn_fwd_splitkv takes the
 * descales explicitly).
 *
 *   q, k, v   device pointers, layout and type as above (read only)
 *   o, lse    device pointers, fp32 outputs (written completely)
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, float* o, float* lse,
                     int B, int H, int Sq, int Sk, int d, float scale, int causal,
                     attn_dtype dtype, void* stream);

/*
 * attn_fwd_ex -- attn_fwd with a choice of output type for O.
 *
 * The pages fix O's type only for one workload (fp32); BF16 is the reduced type they list
 * for the attention kernels next to FP8 ("Inside FlashAttention-3", section 7.3, BF16 / FP8
 * support), here for the output, whose bytes it halves.
 *
 * out_dtype ATTN_F32 is attn_fwd.  ATTN_BF16 writes O as bfloat16 bit patterns (uint16,
 * [B,H,Sq,d]): the same fp32 values attn_fwd computes, each rounded to the nearest bf16
 * (ties to even) at the write-back, which halves the bytes O takes.  lse stays fp32.
 * Other output types return ATTN_ERR_UNSUPPORTED.  Everything else as for attn_fwd.
 */
attn_status attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int Sq, int Sk, int d, float scale, int causal,
                        attn_dtype dtype, attn_dtype out_dtype, void* stream);

/*
 * attn_fwd_varlen -- attn_fwd over a ragged batch: B sequences of different lengths
 * packed without padding (variable-length sequences handled as ragged tensors, as the
 * page "Inside FlashAttention-3", section 7.2, lists for the production integration).
 *
 * Layout (head-major, packed): Q is [H, total_q, d], K and V are [H, total_k, d], O is
 * [H, total_q, d] fp32 and lse is [H, total_q] fp32, all contiguous.  Sequence b owns the
 * query rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) and the key rows
 * [cu_seqlens_k[b], cu_seqlens_k[b+1]) of every head and attends only to its own keys:
 * for each sequence the result is that of attn_fwd with B = 1, Sq = its query count and
 * Sk = its key count (the causal mask aligned to that sequence's bottom-right corner; a
 * sequence with queries but no keys gets O = 0 and lse = -inf on its rows).
 *
 *   cu_seqlens_q, cu_seqlens_k  device pointers to int32 [B+1] (4-byte aligned):
 *                 non-decreasing offsets from 0 to total_q / total_k, each length at
 *                 most max_seqlen_q / max_seqlen_k.  The kernel reads them; the host
 *                 cannot check them without synchronising, which the library never
 *                 does.  Offsets are clamped to [0, total] and lengths to
 *                 [0, max_seqlen] on the device, so entries that break the contract can
 *                 never make a kernel address outside the buffers; they give
 *                 unspecified results.  Rows that no sequence covers are not written.
 *   max_seqlen_q, max_seqlen_k  bounds of the lengths, >= 1; the launch has
 *                 B * H * ceil(max_seqlen_q / 128) four-wavefront workgroups, and those
 *                 past the end of their sequence exit at once.
 *   total_q, total_k  rows per head of Q (and O) and of K / V, >= 1
 * Everything else as for attn_fwd (all dtypes and head dims; fp8 codes used as they
 * are).  The launch is the plain kernel instance of attn_fwd for (d, dtype), the one
 * attn_kernel_name reports for a non-causal call.
 */
attn_status attn_fwd_varlen(const void* q, const void* k, const void* v, float* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            int B, int H, int max_seqlen_q, int max_seqlen_k,
                            int total_q, int total_k, int d, float scale, int causal,
                            attn_dtype dtype, void* stream);

/*
 * attn_splitkv_workspace_bytes -- bytes of the workspace attn_fwd_splitkv writes and
 * attn_merge reads for this shape, or 0 if an argument is out of range.
 *
 * Workspace layout (all fp32, each section starting at a multiple of 256 bytes from
 * the workspace base), with R = B*H*Sq rows and n = num_splits:
 *     m [n][B][H][Sq]   the chunk's softmax reference in natural-log units (-inf: empty)
 *     l [n][B][H][Sq]   sum over the chunk of exp(S - m)
 *     u [n][B][H][Sq][d] sum over the chunk of exp(S - m) * v * v_descale (not divided by l)
 * A chunk state is defined up to its reference: (m + t, l e^-t, u e^-t) is the same state
 * and merges to the same result.  m is the chunk maximum of the scaled scores or lags it:
 * the kernel moves its reference lazily, so m >= max - lag with lag = (log2(448) - 4) ln 2
 * (about 3.33) for FP8 inputs (the 2^4-scaled probabilities stay at or below E4M3's
 * largest value, 448), 8 ln 2 for fp32 inputs and 33 ln 2 (about 22.9) for bf16 inputs
 * (the bf16 key sweep re-references only when a probability would pass 2^33).  A chunk
 * that fits one key tile stores its exact maximum.  m + ln l (the chunk's log-sum-exp) and u / l (its
 * normalised weighted average) do not depend on that choice.  (The split-K section of
 * "AI 大模型之 FlashAttention_02", engineering practice, asks the interface to state this
 * local-statistics layout: axis, per-chunk ownership and merge operator.)
 */
size_t attn_splitkv_workspace_bytes(int B, int H, int Sq, int d, int num_splits);

/*
 * attn_splitkv_num_splits -- a split count for attn_fwd_splitkv chosen from the shape
 * (the split-K section of "AI 大模型之 FlashAttention_02" asks for a choice that follows
 * the shape, since the extra state write-back and merge launch can cancel the gain for
 * short sequences).  Returns 1 when splitting does not pay -- the unsplit grid of
 * B*H*ceil(Sq/128) workgroups already covers the device's CUs, or Sk < 2048 -- else the
 * largest power of two n <= 64 that keeps B*H*ceil(Sq/128)*n within the CU count and every
 * chunk at >= 1024 keys.  Depends on the current device's CU count (a cached HIP query;
 * 1 without a device).  0 if an argument is out of range (as attn_fwd would refuse it).
 */
int attn_splitkv_num_splits(int B, int H, int Sq, int Sk, int d, attn_dtype dtype);

/*
 * attn_fwd_splitkv -- local softmax states of an n-way split of the keys.
 *
 * The key axis is cut into n chunks of C = ceil(Sk / n) keys: chunk s covers keys
 * [s*C, min(Sk, (s+1)*C)); chunks past the end are empty and get the neutral state
 * (m = -inf, l = 0, u = 0).  Each chunk's (m, l, u) is written to the workspace as
 * laid out above (the split-K scheme and worked example of "AI 大模型之
 * FlashAttention_02", section "Engineering practice: reduction along keys vs. along
 * queries").  Combine with attn_merge.
 *
 *   ws, ws_bytes          device workspace and its size in bytes (>= the size above)
 *   num_splits            n, 1 <= n <= ATTN_MAX_SPLITS
 *   q_descale, k_descale  fp32 factors applied to the scores: S = scale*qd*kd*(Q K^T)
 *   v_descale             fp32 factor applied to V (it ends up in u)
 *   (use 1.0 for all three unless the inputs are scaled FP8 codes)
 */
attn_status attn_fwd_splitkv(const void* q, const void* k, const void* v,
                             void* ws, size_t ws_bytes, int num_splits,
                             int B, int H, int Sq, int Sk, int d, float scale, int causal,
                             attn_dtype dtype, float q_descale, float k_descale,
                             float v_descale, void* stream);

/*
 * attn_merge -- combine the n chunk states of a workspace into O and lse.
 *
 * With M = max_s m_s and w_s = exp(m_s - M) (0 for an empty chunk):
 * L = sum_s w_s l_s, O = sum_s w_s u_s / L, lse = M + ln L; a row whose chunks are all
 * empty gets O = 0, lse = -inf.  This is the merge of the split-K section of
 * "AI 大模型之 FlashAttention_02" (each chunk rescaled to the global maximum before
 * summing, normalised once).
 *
 *   ws, ws_bytes   workspace written by attn_fwd_splitkv with the same shape and n
 *   o, lse         device pointers, fp32 outputs [B,H,Sq,d] and [B,H,Sq]
 */
attn_status attn_merge(const void* ws, size_t ws_bytes, int num_splits, float* o, float* lse,
                       int B, int H, int Sq, int d, void* stream);

/*
 * attn_fwd_splitkv_noalloc -- attn_fwd_splitkv followed by attn_merge in one call, with
 * the chunk states in a workspace the library owns: the call allocates nothing.
 *
 * For callers that cannot allocate device memory -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  The workspace is a static device array
 * of ATTN_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until the
 * process ends; its address on a GPU is looked up once, on the first call with that GPU
 * current.  Every state entry is written by the split launch before the merge launch
 * reads it, so nothing is cleared between calls.
 *
 *   q, k, v, num_splits, B, H, Sq, Sk, d, scale, causal, dtype, descales
 *                  as for attn_fwd_splitkv
 *   o, lse         device pointers, fp32 outputs [B,H,Sq,d] and [B,H,Sq], as for attn_merge
 * The result is that of attn_fwd_splitkv + attn_merge with the same arguments (the same
 * two launches, on `stream`).  Returns ATTN_ERR_WORKSPACE, before anything is launched,
 * when attn_splitkv_workspace_bytes(B, H, Sq, d, num_splits) exceeds
 * ATTN_NOALLOC_SCRATCH_BYTES, and ATTN_ERR_HIP if the array's address cannot be found.
 * Calls on one GPU share its one array: calls that overlap on the same GPU (other streams,
 * other threads) race and give wrong results; calls ordered on one stream do not.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
attn_status attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, float* o,
                                     float* lse, int num_splits, int B, int H, int Sq, int Sk,
                                     int d, float scale, int causal, attn_dtype dtype,
                                     float q_descale, float k_descale, float v_descale,
                                     void* stream);

/*
 * attn_bwd_workspace_bytes -- bytes of the workspace attn_bwd needs for this shape, or 0
 * if an argument is out of range.  Layout (each section at a multiple of 256 bytes from
 * the base), R = B*H*Sq rows: dO rounded to bf16 [R][d], D = sum_d dO*O [R] (fp32), lse
 * in log2 units [R] (fp32); causal only, the second-half partial dK and dV [B*H][L*128][d]
 * (fp32) of the L long key tiles (those whose causal sweep covers more than a third of the
 * query rows) and the second-half partial dQ [B*H][M*128][d] (fp32) of the M long query
 * tiles (the last ones, whose sweep covers more than a third of the longest one's keys),
 * which attn_bwd may split between two workgroups.  Contents are scratch.
 */
size_t attn_bwd_workspace_bytes(int B, int H, int Sq, int Sk, int d, int causal);

/*
 * attn_bwd -- gradients of the forward above with respect to Q, K and V.
 *
 * Given the forward's inputs, its outputs O and lse (from attn_fwd with the same
 * arguments) and dO = dL/dO, writes dQ, dK, dV for O = softmax(scale * Q K^T + mask) V:
 *     P = exp(scale * Q K^T - lse) (0 where masked),  dV = P^T dO,  dP = dO V^T,
 *     dS = P * (dP - D) with D_i = sum_d dO_id O_id,  dQ = scale * dS K,  dK = scale * dS^T Q.
 * The probabilities are recomputed from lse, never stored.  dK and dV sum over the
 * queries and dQ over the keys, each inside one workgroup: no atomics, and the result
 * does not depend on timing ("AI 大模型之 FlashAttention_02", section "Training and
 * deployment: backward consistency of split and reduction": the backward reduces across
 * queries, the other direction from the forward's split).  Rows with no visible key
 * (lse = -inf) get dQ = 0 and contribute nothing.
 *
 *   q, k, v      device pointers, [B,H,Sq,d], [B,H,Sk,d], [B,H,Sk,d], bf16 (dtype ATTN_BF16)
 *   o, dout      device pointers, fp32 [B,H,Sq,d]: forward output and upstream gradient
 *   lse          device pointer, fp32 [B,H,Sq]: forward log-sum-exp (natural log)
 *   dq, dk, dv   device pointers, fp32 outputs [B,H,Sq,d], [B,H,Sk,d], [B,H,Sk,d]
 *   ws, ws_bytes device workspace of at least attn_bwd_workspace_bytes(B, H, Sq, Sk, d, causal)
 *   scale, causal as for attn_fwd
 * Supported: dtype ATTN_BF16 with d = 64, 128 or 256 (else ATTN_ERR_UNSUPPORTED).  All
 * pointers 16-byte aligned, buffers contiguous and not overlapping.  dO is used rounded
 * to bf16, and P and dS are rounded to bf16 as operands of the products (fp32
 * accumulation).  Asynchronous on `stream` (three launches, four when long causal query
 * tiles are split); the library allocates nothing.  Errors are returned before any
 * launch.
 */
attn_status attn_bwd(const void* q, const void* k, const void* v, const float* o,
                     const float* dout, const float* lse, float* dq, float* dk, float* dv,
                     void* ws, size_t ws_bytes, int B, int H, int Sq, int Sk, int d,
                     float scale, int causal, attn_dtype dtype, void* stream);

/* Name of a kernel attn_bwd launches: which = 0 prologue, 1 dK/dV, 2 dQ (whose last
 * workgroups also add the halves of split key tiles), 3 the combine pass of split query
 * tiles ("unsupported" if none). */
const char* attn_bwd_kernel_name(int d, attn_dtype dtype, int which);

/*
 * Launch plan queries.  num_splits = 0 describes attn_fwd; num_splits >= 1 describes
 * attn_fwd_splitkv with that many chunks.  A call launches one four-wavefront workgroup
 * per 128 query rows (times num_splits), except causal bf16 calls with d <= 128 whose
 * tiles outnumber the CUs but whose tile pairs fit one workgroup per CU: those launch one
 * eight-wavefront workgroup per pair of 128-row tiles (t, last - t), 256 query rows.
 * (Grids of at most one tile per CU launch eight-wavefront workgroups of 128 query rows
 * whose two halves split the keys, with the same count.)  Plans depend on the current
 * device's CU count (a HIP query) and on a plan stored for the shape by attn_tune or
 * attn_plan_set, if any.
 */
/* Query rows per workgroup, or 0 if an argument is out of range. */
int attn_block_m(int B, int H, int Sq, int Sk, int d, int causal, attn_dtype dtype,
                 int num_splits);

/* Keys per tile of the key sweep of the four-wavefront kernel for (d, dtype), or 0; for
 * bf16 with d = 64 it is the tile of sweeps of at most 4096 keys (32), longer sweeps use
 * 64-key tiles (attn_kernel_name names the instance a shape runs). */
int attn_block_n(int d, attn_dtype dtype);

/* Workgroups of the launch: B * H * ceil(Sq / block_m) * max(1, num_splits), or -1. */
int64_t attn_num_workgroups(int B, int H, int Sq, int Sk, int d, int causal, attn_dtype dtype,
                            int num_splits);

/* Name of the kernel instance the call launches under the plan in effect (static string;
 * "unsupported" if none): the real kernel name a measurement records with its software
 * versions ("AI 大模型之 FlashAttention_02", section "Experiment code and timing
 * discipline").  The head group of a plan (attn_plan_get) does not change the instance. */
const char* attn_kernel_name(int B, int H, int Sq, int Sk, int d, int causal, attn_dtype dtype,
                             int num_splits);

/*
 * Shape-keyed tuning ("Inside FlashAttention-3", section 7.1 Kernel Tuning: benchmark the
 * candidate configurations once and keep the best for later calls; "AI 大模型之
 * FlashAttention_02", section 3.3: the best block configuration differs from shape to
 * shape, and the choice must stay reproducible).
 *
 * A launch plan of attn_fwd / attn_fwd_ex is an integer
 *     plan = schedule + 4 * log2(head_group)
 * schedule 0: one workgroup per 128-row query tile (causal: longest sweeps first);
 *          1: (causal) workgroups i and i + grid/2 get complementary query tiles;
 *          2: (causal bf16, d <= 128) one workgroup per pair of tiles (t, last - t);
 *          3: (bf16 d <= 128, fp8 d = 128) two wavefront groups per workgroup splitting each
 *             tile's keys;
 * head_group (1..64, dividing B*H; schedules 0 and 3 only, else 1): heads whose query tiles
 * are scheduled together on one XCD.  Every plan computes the same attention; schedules
 * differ in rounding order only (3 and 2 merge two partial states).  Without a stored plan
 * a fixed rule picks one (attn_plan_get reports it).
 *
 * Plans are kept per process, keyed by (device, its CU count, dtype, d, causal, B, H, Sq,
 * Sk); stored split counts by the same key without causal.  The table is thread-safe; an
 * empty table costs attn_fwd nothing.
 */

/*
 * attn_tune -- SYNCHRONOUS: times every legal plan of attn_fwd for this shape (`reps`
 * launches each on `stream`, after two untimed ones; median of HIP-event durations),
 * stores the winner for the shape, writes its id to *plan (if plan is not NULL), leaves the
 * winner's O and lse in o / lse and waits for `stream`.  Arguments as for attn_fwd, plus
 * reps in [1, 1000].  The winner is the fastest median, unless it beats the rule's plan by
 * less than 2 %, in which case the rule's plan stays (deterministic for given timings; the
 * margin keeps timing noise from flipping the choice between runs).  Call it before the
 * timed or captured region, never inside a graph capture.
 */
attn_status attn_tune(const void* q, const void* k, const void* v, float* o, float* lse,
                      int B, int H, int Sq, int Sk, int d, float scale, int causal,
                      attn_dtype dtype, int reps, int* plan, void* stream);

/*
 * attn_tune_splitkv -- SYNCHRONOUS: times attn_fwd_splitkv + attn_merge for the split
 * counts 1, 2, 4, ..., 64 (and attn_splitkv_num_splits' rule), with the chunk states in the
 * static array of attn_fwd_splitkv_noalloc, stores the winner (same rule as attn_tune), which
 * attn_splitkv_num_splits returns from then on for (B, H, Sq, Sk, d, dtype), writes it to
 * *num_splits (if not NULL) and leaves its O and lse in o / lse.  Counts whose states exceed
 * ATTN_NOALLOC_SCRATCH_BYTES are not tried (ATTN_ERR_WORKSPACE if the rule's own count does
 * not fit).  Arguments as for attn_fwd_splitkv_noalloc, plus reps in [1, 1000].
 */
attn_status attn_tune_splitkv(const void* q, const void* k, const void* v, float* o, float* lse,
                              int B, int H, int Sq, int Sk, int d, float scale, int causal,
                              attn_dtype dtype, float q_descale, float k_descale,
                              float v_descale, int reps, int* num_splits, void* stream);

/* The plan attn_fwd uses for this shape: the stored one, else the rule's; -1 if an argument
 * is out of range.  With attn_plan_set, a plan chosen in one run can be reused in another. */
int attn_plan_get(int B, int H, int Sq, int Sk, int d, int causal, attn_dtype dtype);

/* Stores `plan` for the shape on the current device (ATTN_ERR_UNSUPPORTED if it is not a
 * legal plan of that shape: unknown schedule for dtype / d / causal, head group not dividing
 * B*H). */
attn_status attn_plan_set(int B, int H, int Sq, int Sk, int d, int causal, attn_dtype dtype,
                          int plan);

/* Forgets every stored plan and split count. */
void attn_plan_clear(void);

/* Human-readable text of a status code (static string). */
const char* attn_status_string(attn_status s);

/* HIP error code of the last failed launch on the calling thread (0 if none). */
int attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */

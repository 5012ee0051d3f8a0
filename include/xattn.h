/*
 * libxattn -- XAttention prefill path for AMD Instinct MI355X (gfx950).
 *
 * The method: "XAttention: Block Sparse Attention with Antidiagonal Scoring"
 * (papercache.org summary).  Section 2.2 ("Threshold Block Selection") defines
 * the problem this library solves: given Q, K in R^{L x d}, block size B,
 * stride S, head dimension d_h and threshold tau, produce a block mask M
 * (Algorithm 1 and the find_blocks equation); section 1 step 3 ("Block Sparse
 * Attention") then computes attention over the selected blocks only.
 *
 * Calls, in the order of the path:
 *   xattn_score          block scores from strided antidiagonal sums
 *   xattn_score_noalloc  the same with a fixed internal scratch (no workspace)
 *   xattn_score_pattern  block scores with another sampling pattern (ablation)
 *   xattn_select         threshold block selection -> mask, index lists
 *   xattn_select_topk    Top-K cut of the same ranking (selection ablation)
 *   xattn_select_topratio  Top-Ratio cut of the same ranking
 *   xattn_score_select   scoring + threshold selection fused (no score matrix)
 *   xattn_sparse_prefill attention over the selected blocks
 *   xattn_dit_attention  dense warm-up steps, then the sparse path (video DiT)
 *   xattn_head_error, xattn_tau_dp  per-head threshold calibration
 *   xattn_full           dense attention (the speed baseline)
 *
 * Conventions for every call:
 *   - Batch 1.  Q and O are [hq][L][d], K and V are [hkv][L][d], contiguous
 *     row-major, dtype = shape->dtype (bf16 or fp32), device memory.  Query
 *     head h reads key/value head h / (hq / hkv).
 *   - Every device buffer (Q, K, V, O, scores, mask, idx, counts, err,
 *     workspace) must start on a 16-byte boundary; a misaligned pointer is
 *     refused with XATTN_EINVAL before any HIP call.
 *   - Every pointer except `tau_host` and `shape` is device memory owned by
 *     the caller.  The library allocates nothing, frees nothing and keeps no
 *     pointer after a call returns.
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls only enqueue
 *     work on that stream and never synchronise the host.
 *   - Arguments are validated before any HIP call.  A call that returns an
 *     error has enqueued nothing, except XATTN_EHIP (a launch failed).
 *     xattn_last_error() returns a thread-local description of the last
 *     error.  No C++ exception crosses this interface.
 *   - Mutable global state is limited to four things:
 *     - per-device caches of the compute-unit count and of two static device
 *       arrays' addresses, each filled once, atomically;
 *     - the work-item counters of the bf16 attention calls: 64 launch slots,
 *       used round robin (see xattn_sparse_prefill);
 *     - the scratch of xattn_score_noalloc;
 *     - the thread-local error string.
 *     Calls are safe to issue from several host threads; calls on one stream
 *     run in order.
 */
#ifndef XATTN_H
#define XATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum xattn_status {
  XATTN_OK = 0,
  XATTN_EINVAL = 1,       /* malformed argument (null pointer, bad shape, tau) */
  XATTN_EUNSUPPORTED = 2, /* well-formed, but outside what the kernels cover */
  XATTN_EWORKSPACE = 3,   /* workspace smaller than xattn_score_workspace_bytes */
  XATTN_EHIP = 4          /* a HIP launch reported an error */
} xattn_status;

typedef enum xattn_dtype { XATTN_FP32 = 0, XATTN_BF16 = 1 } xattn_dtype;

typedef struct xattn_shape {
  int32_t hq;     /* query heads, >= 1 */
  int32_t hkv;    /* key/value heads, >= 1, hq % hkv == 0 */
  int32_t L;      /* tokens, >= 1 */
  int32_t d;      /* head dimension */
  int32_t dtype;  /* xattn_dtype of Q, K, V and O */
  int32_t causal; /* 1: token i attends to keys j <= i; 0: bidirectional */
} xattn_shape;

/* Bytes of device workspace xattn_score needs for this shape (0 if none).
 * Returns 0 as well for arguments xattn_score would reject. */
size_t xattn_score_workspace_bytes(const xattn_shape* shape, int32_t S, int32_t B);

/*
 * Block scores (Algorithm 1 and section 2.1 "antidiagonal selection").
 * For query head h, the stride-S reshape pairs query row R*S+a with key row
 * c*S+S-1-a, so entry (R, c) of Q_reshaped K_reshaped^T is the sum of the
 * antidiagonal of the SxS tile (R, c) of Q K^T.  Each reshaped row R gets a
 * softmax over the L/S columns at scale 1/sqrt(d*S); when causal, columns
 * c > R are excluded.  The block score of (query block qb, key block kb) is
 * the sum of those probabilities over the (B/S)x(B/S) tile divided by B/S,
 * so every query-block row sums to 1.
 *
 *   scores     out, fp32 [hq][NB][NB], NB = L / B.  Fully overwritten;
 *              entries kb > qb are 0 when causal.
 *   workspace  device scratch of at least xattn_score_workspace_bytes().
 * Requires L % B == 0 and B % S == 0 (else XATTN_EINVAL).  bf16 kernels
 * cover d in {64, 128}, B/S in {4, 8, 16, 32} and L * d * 2 < 2^31 bytes per
 * head; fp32 kernels cover d <= 1024 and B/S <= 256 (else
 * XATTN_EUNSUPPORTED).
 */
xattn_status xattn_score(const xattn_shape* shape, const void* Q, const void* K,
                         int32_t S, int32_t B, float* scores, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * xattn_score without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  The scoring partials live in a fixed device array
 * of XATTN_SCORE_SCRATCH_BYTES (64 MiB) inside the library, one copy on every
 * GPU the library runs on, held until the process ends; the call allocates
 * and frees nothing.  A shape whose xattn_score_workspace_bytes() exceeds it
 * is refused with XATTN_EWORKSPACE before any device work (e.g. 32 query
 * heads at L = 16384, S = 8, B = 128 need 50 MiB and fit; L = 32768 does not).
 * The array keeps the last call's contents; nothing needs clearing, since a
 * call rewrites every entry it reads.  All calls on one GPU share it: calls
 * that overlap in time on one GPU (other streams, or other host threads
 * without ordering) race and may return wrong scores; calls ordered on one
 * stream are safe.  Scores are bit-identical to xattn_score's.  Arguments,
 * outputs and other errors as xattn_score.
 */
#define XATTN_SCORE_SCRATCH_BYTES ((size_t)64 << 20)
xattn_status xattn_score_noalloc(const xattn_shape* shape, const void* Q, const void* K,
                                 int32_t S, int32_t B, float* scores, void* stream);

/*
 * Block scores with another sampling pattern inside each SxS tile: the
 * pattern-geometry ablation (chapterpal.com Knowl 9, "Pattern Geometry":
 * antidiagonal vs. diagonal vs. random sampling at the same stride;
 * papercache.org summary, ablation "effectiveness of the antidiagonal
 * pattern").  The pages name the patterns without defining them; here a
 * pattern pairs query sub-row a of each reshaped row with key sub-row
 * phase_host[a] of each reshaped column:
 *   C[R][c] = sum_a <Q[R*S + a], K[c*S + phase_host[a]]>
 * and everything after the product is as xattn_score.  phase_host[a] = S-1-a
 * is xattn_score itself, phase_host[a] = a the diagonal pattern, a random
 * permutation (drawn by the caller) the random pattern.
 *
 *   phase_host  in, HOST array of S int32: a permutation of 0 .. S-1
 *               (else XATTN_EINVAL); S <= 64 (else XATTN_EUNSUPPORTED)
 * Other arguments, workspace (xattn_score_workspace_bytes), outputs and
 * errors as xattn_score.
 */
xattn_status xattn_score_pattern(const xattn_shape* shape, const void* Q, const void* K,
                                 int32_t S, int32_t B, const int32_t* phase_host, float* scores,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Threshold block selection: find_blocks(A, tau) of section 2.2, per (head,
 * query block), over the valid key blocks (kb <= qb when causal, all NB
 * otherwise).  Blocks are ranked by score, highest first, lower kb first on
 * equal scores; the selection is the shortest prefix whose score sum
 * (accumulated in float64) is >= tau[h].  tau[h] == 1, or a tau the prefix
 * sums never reach, selects every valid block.
 *
 *   scores    in, fp32 [hq][NB][NB] (as written by xattn_score)
 *   tau_host  in, HOST array of hq floats, each in (0, 1] (else XATTN_EINVAL)
 *   mask      out, uint64 [hq][NB][(NB+63)/64]: bit kb%64 of word kb/64
 *   idx       out, int32 [hq][NB][NB]: selected kb in ascending order, then -1
 *   counts    out, int32 [hq][NB]: number of selected blocks (>= 1)
 * Covers NB <= 4096 and hq <= 128 (else XATTN_EUNSUPPORTED).
 */
xattn_status xattn_select(int32_t hq, int32_t NB, int32_t causal, const float* scores,
                          const float* tau_host, uint64_t* mask, int32_t* idx,
                          int32_t* counts, void* stream);

/*
 * Fixed-count cut rules compared with the threshold rule in the ablation on
 * block selection strategies (chapterpal.com Knowl 9, "Selection Strategy":
 * Top-K with K = 8192 tokens, Top-Ratio with ratio 27%; papercache.org
 * summary, ablation "block selection strategy").  The pages name the rules
 * without defining them; here both cut the ranking of xattn_select (score
 * descending, lower kb first on ties) at a fixed count, clamped to
 * [1, valid blocks]:
 *   xattn_select_topk      k_blocks blocks (K tokens / B), k_blocks >= 1
 *   xattn_select_topratio  floor(ratio * valid + 0.5) blocks, evaluated in
 *                          float64, ratio in (0, 1]
 * Arguments, outputs, limits and errors otherwise as xattn_select
 * (no per-head tau; hq is not limited to 128).
 */
xattn_status xattn_select_topk(int32_t hq, int32_t NB, int32_t causal, const float* scores,
                               int32_t k_blocks, uint64_t* mask, int32_t* idx, int32_t* counts,
                               void* stream);
xattn_status xattn_select_topratio(int32_t hq, int32_t NB, int32_t causal, const float* scores,
                                   float ratio, uint64_t* mask, int32_t* idx, int32_t* counts,
                                   void* stream);

/*
 * Fused scoring + threshold selection: xattn_score followed by xattn_select
 * (tau per head, antidiagonal pattern) in one call whose block scores never
 * reach memory -- the per-query-block finishing of the scores and the
 * ranking/cut run in one kernel.  Results are bit-identical to the two calls.
 * bf16 only (fp32: XATTN_EUNSUPPORTED).  The workspace is
 * xattn_score_workspace_bytes(shape, S, B) bytes; arguments, outputs and
 * errors otherwise as xattn_score and xattn_select.
 */
xattn_status xattn_score_select(const xattn_shape* shape, const void* Q, const void* K, int32_t S,
                                int32_t B, const float* tau_host, uint64_t* mask, int32_t* idx,
                                int32_t* counts, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * Attention of one layer at one denoising step of a video diffusion
 * transformer under the full-attention warm-up policy (chapterpal.com
 * Knowl 4, "Full-Attention Denoising Warmup"; papercache.org summary, video
 * generation experiment): steps 0 .. warmup_steps-1 (the pages: the first 5
 * of 50) run dense attention (xattn_full); later steps run
 * xattn_score_select with tau_host and then xattn_sparse_prefill.
 *
 *   step, warmup_steps  >= 0 (else XATTN_EINVAL); step counts from 0
 *   workspace           device, xattn_dit_workspace_bytes(shape, S, B) bytes:
 *                       scoring partials, then mask, idx and counts of the
 *                       selection (left there after a sparse step); unused
 *                       (may be NULL) on warm-up steps
 * Other arguments and errors as xattn_full / xattn_score_select /
 * xattn_sparse_prefill (bf16 only on sparse steps).
 */
size_t xattn_dit_workspace_bytes(const xattn_shape* shape, int32_t S, int32_t B);
xattn_status xattn_dit_attention(const xattn_shape* shape, const void* Q, const void* K,
                                 const void* V, int32_t S, int32_t B, const float* tau_host,
                                 int32_t step, int32_t warmup_steps, void* O, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * Minimum threshold prediction (section 2.3; chapterpal.com Knowl 3): per-head
 * thresholds by dynamic programming over threshold-reduction steps, each step
 * multiplying a head's threshold by 0.9.  The pages score a configuration by
 * downstream model accuracy; these calls use a proxy computed on the device,
 * the relative squared error of a head's sparse output against its dense
 * output, and a host DP that is exact for that additive proxy.
 *
 * xattn_head_error: err[h] = sum (O_sparse - O_dense)^2 / sum O_dense^2 over
 *   head h's [L][d] output (0 if O_dense is 0), float64, deterministic.
 *   shape gives hq, L, d and dtype (hkv and causal are not used); O_sparse,
 *   O_dense: device [hq][L][d], 16-byte aligned; err: device, hq doubles.
 *
 * xattn_tau_dp (host only, no device work): err_host[h*(levels+1) + k] is head
 *   h's error after k steps (threshold tau0 * 0.9^k), k = 0 .. levels.
 *   Exactly `steps` steps (0 .. hq*levels, else XATTN_EINVAL) are distributed
 *   to maximise minus the summed error; D[h][m] is the best value over heads
 *   0 .. h-1 with m steps (levels = 1 is the printed recurrence
 *   D[h][m] = max(D[h-1][m], P(h, m))); ties keep the smaller level for the
 *   later head.  Writes level_out[hq] (host) and, if non-NULL, *best_out.
 *   Tables beyond 2^26 entries: XATTN_EUNSUPPORTED.
 */
xattn_status xattn_head_error(const xattn_shape* shape, const void* O_sparse, const void* O_dense,
                              double* err, void* stream);
xattn_status xattn_tau_dp(int32_t hq, int32_t levels, const double* err_host, int32_t steps,
                          int32_t* level_out, double* best_out);

/*
 * Block-sparse attention (section 1, step 3): for query block qb of head h,
 * token i attends to the keys of the blocks idx[h][qb][0 .. counts[h][qb]),
 * intersected with j <= i when causal; softmax at scale 1/sqrt(d) over those
 * keys only, applied to V.
 *
 *   idx, counts  in, as written by xattn_select.  Entries outside [0, NB)
 *                and, when causal, entries > qb are ignored; counts are
 *                clamped to [0, NB].  The list is a set of blocks: a repeated
 *                entry counts once and blocks are visited in ascending
 *                order.  A row with no key gets O = 0.
 *   O            out, [hq][L][d] in the input dtype, fully overwritten.
 * Requires L % B == 0.  bf16 kernels cover d in {64, 128}, B in {64, 128},
 * and NB up to what fits in one CU's LDS beside the K/V tiles (B = 128,
 * d = 128: NB <= 7488, i.e. L <= 958464; more: XATTN_EUNSUPPORTED); fp32
 * kernels cover d in {32, 64, 128}, B <= 256, and NB whose block bitmap fits
 * in LDS beside the fp32 tiles (else XATTN_EUNSUPPORTED).
 * Concurrency: for bf16 with NB <= 16 B (index rows of at most four entries
 * per thread), the call runs one persistent work-group per CU that takes
 * work items from counters in a static device array of 64 launch slots,
 * used round robin (shared with xattn_full).  Calls on one GPU may run
 * concurrently on different streams as long as fewer than 64 of them are in
 * flight at once.  A captured graph replays the slot it was captured with,
 * so two replays of one graph must not overlap.
 */
xattn_status xattn_sparse_prefill(const xattn_shape* shape, const void* Q, const void* K,
                                  const void* V, int32_t B, const int32_t* idx,
                                  const int32_t* counts, void* O, void* stream);

/*
 * Dense attention softmax(Q K^T / sqrt(d)) V (causal if shape->causal): the
 * exact attention the sparse path is measured against.  The pages' speed
 * baseline is dense FlashAttention (papercache.org summary, section A4
 * "baseline models": FlashAttention run through FlashInfer; chapterpal.com
 * Knowl 6, "Prefill Acceleration and End-to-End Speedup", quotes the
 * attention speedup against it); this call is that baseline on the same
 * hardware, sharing the tiles and softmax of xattn_sparse_prefill with every
 * causal-visible key block visited.
 *
 *   O  out, [hq][L][d] in the input dtype, fully overwritten.
 * bf16 kernels need L % 64 == 0, d in {64, 128} and L * d * 2 < 2^31 bytes
 * per head; fp32 kernels cover d in {32, 64, 128} (else XATTN_EUNSUPPORTED).
 * Concurrency: in bf16 the call runs the persistent kernel of
 * xattn_sparse_prefill and shares its 64 launch slots, with the same limit
 * on calls in flight at once.
 */
xattn_status xattn_full(const xattn_shape* shape, const void* Q, const void* K,
                        const void* V, void* O, void* stream);

const char* xattn_status_str(xattn_status status);
const char* xattn_last_error(void);
int32_t xattn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* XATTN_H */

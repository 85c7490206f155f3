/*
 * lrhead.h — C ABI of the MI355X (gfx950) low-rank draft LM head.
 *
 * The method: "EAGLE-4" (yuxiaoba.github.io/tech/en/eagle-4), section
 * "Retrieve vocabulary candidates cheaply, then score them exactly". A
 * low-rank head over the whole vocabulary retrieves candidate tokens for each
 * draft row; only those candidates then get their exact logits from the
 * original full-rank head. The alphasignal news page on EAGLE-4 (section
 * "Runtime-sized speculation", item "Low-rank candidate head") adds that the
 * head factors token prediction into smaller matrices. In symbols, for a
 * draft row h (length d):
 *
 *     z      = Q . h            Q is r x d           (rank-r down-projection)
 *     s[v]   = P[v,:] . z       P is V x r           (every vocabulary row v)
 *     C      = first k ids under: higher s first, lower id on equal s
 *     logit  = W[C[j],:] . h    W is V x d           (exact, full rank)
 *
 * The full head that the method replaces (the same page, profile of the
 * draft forward in which the full head takes most of the time) is
 * L = W . h over all V rows; fullhead_topk computes it as the baseline.
 *
 * Conventions for every call below
 * --------------------------------
 *  - Matrices are row-major and contiguous. Q: r x d, P: V x r, W: V x d,
 *    H: B x d (one draft row per matrix row), idx / score / logits: B x k.
 *  - Element type of Q, P, W and H is the handle's dtype: LRHEAD_BF16
 *    (bfloat16 bit patterns) or LRHEAD_FP32 (IEEE float). Accumulation is
 *    always fp32. z is stored in the handle's dtype, rounded to nearest-even
 *    from the fp32 accumulator. idx is int32; score and logits are fp32.
 *  - Every pointer except `stream` and the handle is a DEVICE pointer and
 *    must be 16-byte aligned. `stream` is a hipStream_t (NULL = the default
 *    stream).
 *  - Calls are asynchronous on `stream`: they validate their arguments on
 *    the host, enqueue kernels and return. They never synchronise and never
 *    allocate device memory. Outputs are valid once the stream reaches them.
 *  - Errors: every call returns LRHEAD_OK (0) or a negative code. Argument
 *    errors are detected on the host before anything is enqueued. A failed
 *    kernel launch returns LRHEAD_EHIP with the HIP text in
 *    lrhead_last_error(). Faults inside kernels surface, as usual in HIP, at
 *    the caller's next synchronisation. Inputs holding NaN or Inf give
 *    undefined ids (the order of the method needs comparable scores).
 *  - B == 0 is valid and enqueues nothing.
 *  - Ownership: Q, P, W and the workspace are borrowed for the lifetime of
 *    the handle; H, idx, score and logits are borrowed until the stream
 *    reaches the call. The handle owns only host memory.
 *  - Calls on one handle share its workspace, so they must be ordered on one
 *    stream. Use one handle (and workspace) per concurrent stream.
 */
#ifndef LRHEAD_H
#define LRHEAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lrhead_s* lrhead_t;

/* Element types of Q, P, W and H. */
#define LRHEAD_BF16 0
#define LRHEAD_FP32 1

/* Return codes. */
#define LRHEAD_OK          0
#define LRHEAD_EINVAL     (-1)  /* null pointer, non-positive size, bad handle   */
#define LRHEAD_ERANGE     (-2)  /* k, B, r or d outside the supported range      */
#define LRHEAD_EDTYPE     (-3)  /* unknown dtype                                 */
#define LRHEAD_EALIGN     (-4)  /* a device pointer is not 16-byte aligned       */
#define LRHEAD_EWORKSPACE (-5)  /* workspace smaller than lrhead_workspace_bytes */
#define LRHEAD_EHIP       (-6)  /* a HIP call failed; see lrhead_last_error()    */
#define LRHEAD_EDEVICE    (-7)  /* current device is not an MI355X (gfx950)      */

/* Supported ranges (checked on the host). */
#define LRHEAD_K_MAX   64       /* candidates per row: 1 <= k <= min(k_max, V)   */
#define LRHEAD_R_MAX   512      /* rank of the low-rank head, multiple of 8      */
#define LRHEAD_D_MAX   65536    /* hidden size, multiple of 8                    */

/*
 * Size in bytes of the device workspace a handle with these shapes needs
 * (z for B_max rows, the per-vocabulary-slice candidate lists and their
 * counters). Pure host arithmetic. Returns 0 when the shapes are invalid.
 */
size_t lrhead_workspace_bytes(int dtype, int64_t V, int64_t d, int64_t r,
                              int64_t B_max, int k_max);

/*
 * Creates a handle over a low-rank head (Q, P) and its full-rank head W
 * ("EAGLE-4", section "Retrieve vocabulary candidates cheaply, then score
 * them exactly": the low-rank head retrieves, the original full-rank head
 * scores). Q: r x d, P: V x r, W: V x d, device pointers in `dtype`.
 * B_max bounds the rows of later calls, k_max (<= 64) their k. `workspace`
 * is a device buffer of at least lrhead_workspace_bytes(...) bytes.
 * Requirements: V >= 1, 8 <= d <= 65536 and 8 <= r <= 512 (both multiples of
 * 8), 1 <= k_max <= min(64, V), B_max >= 1. On success *out receives the
 * handle. Fails with LRHEAD_EDEVICE when the current device is not gfx950.
 */
int lrhead_create(lrhead_t* out, int dtype, int64_t V, int64_t d, int64_t r,
                  const void* Q, const void* P, const void* W,
                  int64_t B_max, int k_max, void* workspace,
                  size_t workspace_bytes);

/*
 * Low-rank candidate retrieval ("EAGLE-4", section "Retrieve vocabulary
 * candidates cheaply, then score them exactly": a low-rank head over the
 * full vocabulary selects candidates; it does not supply final
 * probabilities). For each row b of H (B x d): z_b = Q.h_b (stored rounded
 * in the handle's dtype), s_b[v] = P[v,:].z_b for all V rows, and
 * idx[b, 0..k) = the k ids with the highest s_b, higher score first, the
 * lower id first on equal scores. score[b, j] = s_b[idx[b, j]] (fp32);
 * `score` may be NULL. Requires 0 <= B <= B_max, 1 <= k <= k_max.
 */
int lrhead_candidates(lrhead_t h, const void* H, int64_t B, int k,
                      int32_t* idx, float* score, void* stream);

/*
 * Exact rescoring of candidates with the original full-rank head ("EAGLE-4",
 * section "Retrieve vocabulary candidates cheaply, then score them exactly":
 * the candidates' exact logits come from the original full-rank head).
 * logits[b, j] = W[idx[b, j], :] . h_b with fp32 accumulation, for B x k
 * pairs; an id outside [0, V) yields NaN for that entry. With idx == NULL
 * the call computes the dense logits of all V rows into logits (B x V) —
 * a test aid, not part of the method's fast path. Requires 0 <= B <= B_max
 * and, with idx, 1 <= k <= k_max.
 */
int fullhead_logits(lrhead_t h, const void* H, int64_t B,
                    const int32_t* idx, int k, float* logits, void* stream);

/*
 * The full-head baseline the low-rank head replaces ("EAGLE-4", section
 * "Retrieve vocabulary candidates cheaply, then score them exactly": the
 * profiled draft forward in which the full head is 65.4% of the time).
 * L_b = W . h_b over all V rows, then the same top-k rule as
 * lrhead_candidates: idx[b, 0..k) and logits[b, j] = L_b[idx[b, j]].
 * Same output contract as lrhead_draft. Requires 0 <= B <= B_max,
 * 1 <= k <= k_max.
 */
int fullhead_topk(lrhead_t h, const void* H, int64_t B, int k,
                  int32_t* idx, float* logits, void* stream);

/*
 * One draft-head call: lrhead_candidates followed by fullhead_logits on its
 * ids (the two stages of "EAGLE-4", section "Retrieve vocabulary candidates
 * cheaply, then score them exactly"), enqueued back to back. `score` may be
 * NULL.
 */
int lrhead_draft(lrhead_t h, const void* H, int64_t B, int k,
                 int32_t* idx, float* score, float* logits, void* stream);

/*
 * lrhead_draft without a handle and without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation). The workspace is a
 * device array inside the library, LRHEAD_STATIC_SCRATCH_MB MiB, one per GPU,
 * held until the process ends; the first call on a device looks its address
 * up (no allocation follows). Arguments as lrhead_create followed by
 * lrhead_draft with B_max = B and k_max = k (Q, P, W, H device pointers in
 * `dtype`; idx, score (may be NULL), logits: B x k). Returns
 * LRHEAD_EWORKSPACE, before anything is enqueued, when the call needs more
 * scratch than the array holds (lrhead_workspace_bytes(dtype, V, d, r, B, k)
 * above LRHEAD_STATIC_SCRATCH_MB MiB; e.g. at V = 151936 the few-row path up
 * to B = 8 fits). Calls on one GPU share the array, so calls that overlap in
 * time on one GPU (different streams, or host threads) race and give wrong
 * results; order them on one stream. Nothing in the array needs clearing:
 * every call writes what it later reads.
 */
#define LRHEAD_STATIC_SCRATCH_MB 64
int lrhead_draft_static(int dtype, int64_t V, int64_t d, int64_t r, const void* Q, const void* P,
                        const void* W, const void* H, int64_t B, int k, int32_t* idx, float* score,
                        float* logits, void* stream);

/*
 * The draft distribution over each node's candidates and the node's branches
 * ("EAGLE-4: One Flexible Drafter for All Batch Sizes and Hardware":
 * section "Retrieve vocabulary candidates cheaply, then score them exactly",
 * the probabilities come from the exact logits; section "Why a draft tree
 * needs a cost model", products of draft probabilities estimate the benefit.
 * "EAGLE-4 Triples Qwen3 Inference Speed by Adapting to Serving Load",
 * section "Runtime-sized speculation": one branch per node drafts a chain,
 * more a tree). For each of the B rows of `logits` / `idx` (device, B x k
 * row-major, as written by lrhead_draft):
 *   probs[b, j] = exp(l_j - m) / sum_i exp(l_i - m), over the row's k
 *   candidates only (the full-vocabulary normaliser would need all V
 *   logits); NaN logits mark empty slots and get 0;
 *   br_idx[b, r], br_prob[b, r] (r < nb): the nb most probable candidates in
 *   order, equal probabilities going to the lower token id; slots past the
 *   existing candidates hold -1 and 0;
 *   br_path[b, r] = parent[b] * br_prob[b, r] (parent may be NULL: 1).
 * Requirements: 1 <= nb <= k <= 64, B >= 0, device pointers, outputs
 * B x k (probs) and B x nb (the rest), fp32 / int32. Needs no handle and no
 * workspace; asynchronous on `stream`.
 */
int lrhead_branch(const float* logits, const int32_t* idx, const float* parent,
                  int64_t B, int k, int nb, float* probs, int32_t* br_idx,
                  float* br_prob, float* br_path, void* stream);

/*
 * Builds a low-rank head from a full-rank one (the pages factor token
 * prediction into smaller matrices, "EAGLE-4 Triples Qwen3 Inference Speed
 * by Adapting to Serving Load", section "Runtime-sized speculation", but do
 * not say how): a randomized range finder with q subspace iterations,
 *   Y = orth(W . omega);  q times: Z = orth(W^T . Y), Y = orth(W . Z);
 *   P = Y (V x r, orthonormal columns),  Q = Y^T . W (r x d),
 * orth() being CholeskyQR2 with fp64 Gram matrices, so P . Q is W projected
 * onto the captured column space (exactly W when W has rank r). With V and
 * d multiples of 8 the W-sized products run on the bf16 matrix cores, each
 * fp32 panel taken as the sum of two bf16 halves (within 2^-17 of it).
 * W: V x d bf16; omega: d x r fp32 (the Gaussian test matrix, supplied by the
 * caller); P: V x r and Q: r x d bf16 outputs; all device pointers, 16-byte
 * aligned, row-major. Requirements: 1 <= r <= min(512, d, V), 0 <= q <= 8,
 * workspace of at least lrhead_factor_workspace_bytes(V, d, r) bytes.
 * Asynchronous on `stream`; it may allocate nothing and synchronises nothing.
 * A Gram matrix that is not positive definite (W of rank below r) gets tiny
 * pivots, and P is then not orthonormal in the missing directions.
 */
size_t lrhead_factor_workspace_bytes(int64_t V, int64_t d, int r);
int lrhead_factor(const void* W, int64_t V, int64_t d, int r, int q,
                  const float* omega, void* P, void* Q, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * Profiling aid: hipEvent_t handles (passed as void*) that later calls on
 * this handle attach to the dispatch of the vocabulary score pass
 * (lrhead_candidates, lrhead_draft, fullhead_topk; for row batches its main
 * GEMM pass): the first records the kernel's start, the second its end, so
 * hipEventElapsedTime gives that kernel's own duration. Pass NULL, NULL to
 * stop. The events are borrowed; recording them is the only effect. Calls
 * with events set must not be captured into a HIP graph.
 */
int lrhead_set_stage_events(lrhead_t h, void* before, void* after);

/* Releases the handle's host memory (never the borrowed device buffers). */
void lrhead_destroy(lrhead_t h);

/* Static text for a return code. */
const char* lrhead_strerror(int code);

/* Detail of the last error on the calling thread (e.g. the HIP error text). */
const char* lrhead_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LRHEAD_H */

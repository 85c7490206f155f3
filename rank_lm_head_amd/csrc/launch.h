// launch.h — host-side launchers of the head's kernels (internal to the
// library; the public interface is include/lrhead.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrh {

// Optional events attached to one kernel's dispatch: they record its start
// and end (the profiling hook of the score pass).
struct Timing {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

#define LRH_LAUNCH(timing, kernel, grid, block, shm, stream, ...)                                    \
  do {                                                                                           \
    if ((timing).start)                                                                          \
      hipExtLaunchKernelGGL(kernel, grid, block, shm, stream, (timing).start, (timing).stop, 0,  \
                            __VA_ARGS__);                                                        \
    else                                                                                         \
      hipLaunchKernelGGL(kernel, grid, block, shm, stream, __VA_ARGS__);                         \
  } while (0)

// Draft calls with up to kRowsMaxB rows, and full-head calls with up to
// kLongB rows, use the streaming kernels of kernels_small.hip (one pass over
// P or W): draft calls of kRowsMinB to kRowsMaxB rows the matrix-core pass
// that keeps the slice lists in registers, smaller ones (and ranks below 32)
// the pass that stages the scores in LDS (2-4 rows on the matrix cores, one
// row and the full head on the vector ALU); larger bf16 batches use the tiled
// matrix-core kernels.
constexpr int kSmallB = 8;
constexpr int kLongB = 4;

// ----------------------------------------------------- kernels_small.hip
// Blocks (= candidate lists per row) of the streaming selection over V rows.
int small_blocks(int64_t V);
// Whether a call with B rows and rank (row length) K takes the streaming path.
bool small_path(int dtype, int64_t B, int64_t K, int64_t V);
bool small_long_path(int dtype, int64_t B, int64_t K, int64_t V);

// Streaming score pass: per block, the small_list_len(k) best of its slice
// for each row, written depth-major (entry j of block x's list at
// part_[row][j][x]), and every score to raw[row][v] (B x V).
constexpr int kSliceList = 4;
int small_list_len(int k);
hipError_t launch_select_small(const void* M, const void* X, int64_t V, int K, int64_t B, int k, float* part_s,
                               int* part_i, float* raw, hipStream_t stream, Timing t = {});
hipError_t launch_select_long(const void* M, const void* X, int64_t V, int K, int64_t B, int k, float* part_s,
                              int* part_i, hipStream_t stream, Timing t = {});
// kRowsMinB to kRowsMaxB draft rows (bf16, power-of-two 32 <= r <= 512):
// the same slice lists from the matrix-core stream, row-major (entry j of
// block x's list for row b at part_[b][x][j]), no raw scores (the merge
// recomputes a slice it needs more of). From 5 rows on it is the faster pass (cold calls at r = 128,
// k = 32: 22.9 against 24.7 us at 8 rows, 21.6 against 21.8 at 4, 20.5
// against 20.0 at 2).
constexpr int kRowsMinB = 5;
constexpr int kRowsMaxB = 64;
bool rows_path(int dtype, int64_t B, int64_t K, int64_t V);
hipError_t launch_select_rows(const void* M, const void* X, int64_t V, int K, int64_t B, int k, float* part_s,
                              int* part_i, hipStream_t stream, Timing t = {});

// ------------------------------------------------------- kernels_b1.hip
// z = round(Q . h) for B <= kDownWideMaxB rows, one block per row of Q (two
// above 48 rows at r <= 256) and group of 8 rows; block 0
// also zeroes nsync completion counters (128 bytes apart) of the next pass,
// and the blocks mark its n_lgs speculative logits "not written".
constexpr int kDownWideMaxB = 64;
hipError_t launch_down_wide(const void* Q, const void* H, int r, int d, int64_t B, void* Z, uint32_t* sync,
                            int nsync, float* lgs, int n_lgs, hipStream_t stream);
// The one-row call in one pass after the down-projection: score stream,
// slice lists, the speculative logit of each slice's best entry, and the
// merge with the remaining logits in the pass's last block.
constexpr int kB1Counters = 9;   // completion counters the pass uses
constexpr int kB1MaxLists = 512; // slice lists of the pass (blocks)
constexpr int kB1MaxList = 4;    // entries per list
int b1_blocks(int64_t V, int n_cu);
bool b1_path(int dtype, int64_t B, int64_t K, int64_t V, int n_cu);
int b1_list_len(int k);
struct B1Args {
  const void* P;
  const void* Z;
  int64_t V;
  int K;             // rank r
  int k;
  int L;             // slice list length, min(4, k)
  const void* W;     // with logits
  const void* H;
  int d;
  uint64_t* keys;    // lists: candidate key of entry j of list x at [j * n + x]
  float* lgs;        // and its exact logit
  float* raw;        // V raw scores (read only when L < k)
  uint32_t* sync;    // kB1Counters counters, zeroed by launch_down_wide
  int n_cu;
  int32_t* idx;
  float* score;      // may be NULL
  float* logits;     // NULL: candidates only
};
hipError_t launch_draft1(const B1Args& a, hipStream_t stream, Timing t = {});

// ------------------------------------------------------ kernels_mfma.hip
// Vocabulary slices of the matrix-core selection pass for B rows over V
// tokens. The same plan sizes the workspace, so it depends only on (B, V).
int plan_vsplit(int64_t B, int64_t V);

// z = round(Q . h) for B rows: Z is B x r in the weight dtype.
hipError_t launch_down(int dtype, const void* Q, const void* H, int r, int d, int64_t B,
                       void* Z, hipStream_t stream);
// The same for bf16 row batches, split over K across blocks: fp32 partial
// sums (down_split_parts(d) x B x r) in `part`, then a reduction in a fixed
// order and the rounding to bf16.
int down_split_parts(int d);
// Adds S partial sums part[s][i] (i < n) in s order and rounds to bf16: Z[i].
hipError_t launch_down_reduce(const float* part, int S, int64_t n, void* Z, hipStream_t stream);
hipError_t launch_down_split(const void* Q, const void* H, int r, int d, int64_t B, void* Z, float* part,
                             hipStream_t stream);

// Per-slice candidate lists of "M . x" for B rows: M is V x K (P or W),
// X is B x K (z or h). Writes part_s / part_i: [B][k][n_vsplit].
hipError_t launch_select(int dtype, const void* M, const void* X, int64_t V, int K, int64_t B,
                         int k, int n_vsplit, float* part_s, int* part_i, hipStream_t stream, Timing t = {});

// Dense logits[b, v] = W[v, :] . h_b for all V (test aid).
hipError_t launch_dense(int dtype, const void* W, const void* H, int64_t V, int d, int64_t B,
                        float* logits, hipStream_t stream);

// ------------------------------------------------------ kernels_gemm.hip
// bf16 row batches (B > kLongB) that the streaming path does not take use
// the matrix-core GEMM with a sampled per-row bound and an exact collect (no
// per-slice lists).
bool batch_path(int dtype, int64_t B);

struct BatchPlan {
  int64_t nvb;      // vocabulary blocks of 256 rows
  int stride;       // sample pass: every stride-th block
  int ns;           // sampled blocks
  int ns_tiles;     // tile maxima per row (ns * 16 <= 2048)
  int64_t ldS;      // row stride of the sparse score array (nvb * 256)
  int NW;           // mask words per row
};
BatchPlan plan_batch(int64_t V, int64_t B, int k);

struct BatchScratch {
  float* tmax;      // B_max x 2048 tile maxima
  float* theta;     // B_max per-row bounds
  uint32_t* mask;   // B_max x NW flags
  float* S;         // B_max x ldS sparse scores
  size_t S_bytes;
};
size_t batch_scratch_bytes(int64_t V, int64_t B_max);
BatchScratch batch_scratch(void* base, int64_t V, int64_t B_max);
// Lets the GEMM kernels use more than 64 KiB of LDS (call once per device).
hipError_t batch_init();
// fp32 products on the GEMM kernel: S[s][n][m] = sum over the s-th of
// `ksplit` shares of K of X[n][k] M[m][k] (M: Mrows x K, X: Xrows x K, bf16,
// K a multiple of 8; S: ksplit x Xrows x Mrows fp32). Call batch_init()
// once per device first.
hipError_t launch_gemm_f32(const uint16_t* M, int64_t Mrows, int K, const uint16_t* X, int64_t Xrows, float* S,
                           int ksplit, hipStream_t stream);
// z = round_bf16(Q . h) for B rows on the GEMM kernel (bf16 only). With
// too few output tiles to fill the GPU, K is split over blocks (about 512 of
// them) whose fp32 partial sums go to `part` (when part_bytes holds them)
// and are added in a fixed order by launch_down_reduce.
hipError_t launch_down_gemm(const void* Q, const void* H, int r, int d, int64_t B, void* Z, float* part,
                            size_t part_bytes, hipStream_t stream);

// The k best of every row of X . M^T (M is V x K, X is B x K, bf16) in
// candidate order to idx / score (score may be NULL). `t` times the main
// GEMM pass.
hipError_t launch_batch_select(const void* M, const void* X, int64_t V, int K, int64_t B, int k,
                               const BatchScratch& w, int32_t* idx, float* score, hipStream_t stream,
                               Timing t = {});

// ----------------------------------------------------- kernels_merge.hip
// Merges n sorted lists of L entries per row (part_[row][entry][list], or
// with `rowmajor` part_[row][list][entry]; n <= 512) into the k best, to
// idx / score (score may be NULL). Lists
// shorter than k (L < k) come with the rows' raw scores (raw[row][v], list p
// holding the best of the slice [V*p/n, V*(p+1)/n)), or, with raw NULL, with
// P (V x K) and Z (B x K), bf16, from which the merge recomputes the scores
// of a slice it needs (lists from the matrix-core stream only); with L == k
// all three may be NULL. With logits != NULL, also writes the winners'
// exact logits W[id] . h_b, with `speculate` starting on the candidates'
// logits while the winners are ranked.
hipError_t launch_merge(int dtype, const float* part_s, const int* part_i, int n, int L, bool rowmajor,
                        const float* raw, const void* P, const void* Z, int K, int64_t V, int64_t B, int k,
                        const void* W, const void* H, int d, int32_t* idx, float* score, float* logits,
                        bool speculate, hipStream_t stream);

// ---------------------------------------------------- kernels_branch.hip
// Softmax of each row's k candidate logits, the nb most probable as
// branches (ties to the lower id) and their path probabilities.
hipError_t launch_branch(const float* logits, const int32_t* idx, const float* parent, int64_t B, int k, int nb,
                         float* probs, int32_t* br_idx, float* br_prob, float* br_path, hipStream_t stream);

// ---------------------------------------------------- kernels_factor.hip
// P (V x r) and Q (r x d), bf16, from W (V x d, bf16) by a randomized range
// finder with q subspace iterations; omega is d x r fp32.
size_t factor_workspace_bytes(int64_t V, int64_t d, int r);
hipError_t launch_factor(const void* W, int64_t V, int64_t d, int r, int q, const float* omega, void* P, void* Q,
                         void* workspace, hipStream_t stream);

// logits[b, j] = W[idx[b, j], :] . h_b (NaN for ids outside [0, V)).
hipError_t launch_rescore(int dtype, const void* W, const void* H, const int32_t* idx, int64_t B,
                          int k, int64_t V, int d, float* logits, hipStream_t stream);

}  // namespace lrh

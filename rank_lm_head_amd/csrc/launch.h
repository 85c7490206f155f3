// launch.h — host-side launchers of the head's kernels (internal to the
// library; the public interface is include/lrhead.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrh {

// Vocabulary slices of the selection pass for B rows over V tokens. The
// same plan sizes the workspace, so it must depend only on (B, V).
int plan_vsplit(int64_t B, int64_t V);

// z = round(Q . h) for B rows: Z is B x r in the weight dtype.
hipError_t launch_down(int dtype, const void* Q, const void* H, int r, int d, int64_t B,
                       void* Z, hipStream_t stream);

// Per-slice candidate lists of "M . x" for B rows: M is V x K (P or W),
// X is B x K (z or h). Writes part_s / part_i: [B][n_vsplit][k].
hipError_t launch_select(int dtype, const void* M, const void* X, int64_t V, int K, int64_t B,
                         int k, int n_vsplit, float* part_s, int* part_i, hipStream_t stream);

// Merges n_parts sorted lists of k per row into idx / score (score may be NULL).
hipError_t launch_merge(const float* part_s, const int* part_i, int n_parts, int64_t B, int k,
                        int32_t* idx, float* score, hipStream_t stream);

// logits[b, j] = W[idx[b, j], :] . h_b (NaN for ids outside [0, V)).
hipError_t launch_rescore(int dtype, const void* W, const void* H, const int32_t* idx, int64_t B,
                          int k, int64_t V, int d, float* logits, hipStream_t stream);

// Dense logits[b, v] = W[v, :] . h_b for all V (test aid).
hipError_t launch_dense(int dtype, const void* W, const void* H, int64_t V, int d, int64_t B,
                        float* logits, hipStream_t stream);

}  // namespace lrh

// kernels_branch.hip — the draft distribution over one node's candidates.
//
// The low-rank stage only selects candidates; their probabilities come from
// the exact logits of the full-rank head ("EAGLE-4: One Flexible Drafter for
// All Batch Sizes and Hardware", section "Retrieve vocabulary candidates
// cheaply, then score them exactly"), and products of draft probabilities
// along a path estimate the benefit of drafting it (same page, section "Why
// a draft tree needs a cost model"). A node keeps its nb most probable
// candidates as branches: nb = 1 drafts a chain, larger nb a tree ("EAGLE-4
// Triples Qwen3 Inference Speed by Adapting to Serving Load", section
// "Runtime-sized speculation").
//
// branch_kernel: one wave per row, lane j holding candidate j (k <= 64).
//   p_j = exp(l_j - m) / sum_i exp(l_i - m) over the candidates that exist
//   (NaN logits mark empty slots and weigh 0), m the largest logit; the
//   normaliser runs over the candidates only. Each candidate's rank among
//   the row's (probability descending, then token id ascending) comes from
//   counting the keys above it (broadcast LDS reads), and ranks below nb are
//   written as branches with their path probability parent * p.
#include "launch.h"
#include "topk.h"

namespace lrh {

constexpr int kBranchWaves = 4;

__global__ void __launch_bounds__(kBranchWaves * kWave) branch_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx, const float* __restrict__ parent,
    int64_t B, int k, int nb, float* __restrict__ probs, int32_t* __restrict__ br_idx,
    float* __restrict__ br_prob, float* __restrict__ br_path) {
  __shared__ uint64_t keys[kBranchWaves][kWave];
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int64_t b = (int64_t)blockIdx.x * kBranchWaves + wave;
  if (b >= B) return;   // whole waves
  const bool in = lane < k;
  const float l = in ? logits[b * k + lane] : __builtin_nanf("");
  const int id = in ? idx[b * k + lane] : kSentinelId;
  const bool valid = !__builtin_isnan(l);
  const uint32_t mk = wave_max_u32(valid ? order_key(l) : 0u);
  const float m = mk ? __uint_as_float(order_key_inv(mk)) : 0.f;
  const float e = valid ? expf(l - m) : 0.f;
  const float s = group_sum<kWave>(e);
  const float p = s > 0.f ? e / s : 0.f;
  if (in) probs[b * k + lane] = p;

  const uint64_t key = valid ? ((uint64_t)order_key(p) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id) : 0ull;
  keys[wave][lane] = key;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const u64x2* k2 = reinterpret_cast<const u64x2*>(keys[wave]);
  int r = 0;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u64x2 a[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) a[q] = k2[16 * h + q];
#pragma unroll
    for (int q = 0; q < 16; ++q) r += (a[q].x > key) + (a[q].y > key);
  }
  const float par = parent ? parent[b] : 1.f;
  const int64_t o = b * nb;
  if (valid && r < nb) {
    br_idx[o + r] = id;
    br_prob[o + r] = p;
    br_path[o + r] = par * p;
  }
  const int nvalid = __popcll(__ballot(valid));
  if (lane >= nvalid && lane < nb) {   // fewer candidates than branches
    br_idx[o + lane] = -1;
    br_prob[o + lane] = 0.f;
    br_path[o + lane] = 0.f;
  }
}

hipError_t launch_branch(const float* logits, const int32_t* idx, const float* parent, int64_t B, int k, int nb,
                         float* probs, int32_t* br_idx, float* br_prob, float* br_path, hipStream_t stream) {
  if (B < 0 || k < 1 || k > kWave || nb < 1 || nb > k) return hipErrorInvalidValue;
  if (B == 0) return hipSuccess;
  const dim3 grid((unsigned)((B + kBranchWaves - 1) / kBranchWaves));
  hipLaunchKernelGGL(branch_kernel, grid, dim3(kBranchWaves * kWave), 0, stream, logits, idx, parent, B, k, nb,
                     probs, br_idx, br_prob, br_path);
  return hipGetLastError();
}

}  // namespace lrh

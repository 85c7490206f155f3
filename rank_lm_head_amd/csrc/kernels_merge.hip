// kernels_merge.hip — the k best of the slice lists, and exact rescoring.
//
// After the score pass every draft row has n sorted lists (one per
// vocabulary slice) of its slice's k best ids. merge_kernel finds the row's
// k best overall and, in the draft-head call, gives them their exact logits
// with the full-rank head ("EAGLE-4", section "Retrieve vocabulary
// candidates cheaply, then score them exactly": the retrieved candidates are
// scored exactly by the original full-rank head).
//
// Merge. Take any bound T that at least k list heads (best entries) reach.
// Then at least k entries reach T, so an entry below T is preceded by k
// others and cannot win, and a list whose head is below T holds no winner.
// Wave 0 finds a T that between k and 64 heads reach (windowed bisection,
// topk.h), the block collects the entries of those active lists that reach
// T (a few k of them), and wave 0 ranks the k best of those.
//
// Rescoring: logit = W[id, :] . h with fp32 accumulation, one wave per
// candidate, every load of the W row and of h issued before the products.
#include "launch.h"
#include "topk.h"

namespace lrh {

constexpr int kMergeWaves = 8;
constexpr int kMergeThreads = kMergeWaves * kWave;
constexpr int kMaxLists = kMergeWaves * kWave;   // heads sorted at once

// ------------------------------------------------------------- row dot
template <typename T>
__device__ __forceinline__ float dot_chunk(u32x4 w, u32x4 h, float acc);
template <>
__device__ __forceinline__ float dot_chunk<uint16_t>(u32x4 w, u32x4 h, float acc) {
  return dot8_bf16(w, h, acc);
}
template <>
__device__ __forceinline__ float dot_chunk<float>(u32x4 w, u32x4 h, float acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) acc = fmaf(__uint_as_float(w[q]), __uint_as_float(h[q]), acc);
  return acc;
}

// w . h over d elements by one wave; every lane returns the sum. Up to 16
// wave loads of each operand are in flight; loads past d read a clamped,
// valid address and are zeroed, so none is predicated.
template <typename T>
__device__ __forceinline__ float wave_row_dot(const T* __restrict__ w, const T* __restrict__ h, int d) {
  constexpr int per = 16 / sizeof(T);
  constexpr int U = 16;
  const int lane = threadIdx.x & 63;
  float acc = 0.f;
  for (int c0 = 0; c0 < d; c0 += U * kWave * per) {
    u32x4 wv[U], hv[U];
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const int c = c0 + (t * kWave + lane) * per;
      const int cc = c < d ? c : d - per;
      wv[t] = load16(w + cc);
      hv[t] = load16(h + cc);
    }
#pragma unroll
    for (int t = 0; t < U; ++t) {
      const bool ok = c0 + (t * kWave + lane) * per < d;
      acc = dot_chunk<T>(ok ? wv[t] : u32x4{0u, 0u, 0u, 0u}, hv[t], acc);
    }
  }
  return group_sum<kWave>(acc);
}

// ------------------------------------------------------------ rescoring
// One wave per (row, candidate) pair; ids outside [0, V) give NaN.
template <typename T>
__global__ void __launch_bounds__(256) rescore_kernel(const T* __restrict__ W, const T* __restrict__ H,
                                                      const int32_t* __restrict__ idx, int64_t npairs, int k,
                                                      int64_t V, int d, float* __restrict__ logits) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t pair = (int64_t)blockIdx.x * 4 + wave;
  if (pair >= npairs) return;
  const int64_t b = pair / k;
  const int32_t v = idx[pair];
  if (v < 0 || v >= V) {
    if (lane == 0) logits[pair] = __builtin_nanf("");
    return;
  }
  const float acc = wave_row_dot<T>(W + (int64_t)v * d, H + b * (int64_t)d, d);
  if (lane == 0) logits[pair] = acc;
}

// ---------------------------------------------------------------- merge
constexpr int kHeadE = kMaxLists / kWave;   // heads per lane of wave 0
constexpr int kCandE = 8;                   // candidates per lane of wave 0
constexpr int kCandSlots = kCandE * kWave;

struct MergeSmem {
  uint64_t cand[kCandSlots];
  uint64_t tmp[kWave];
  int active[kWave];
  float top_s[kWave];
  int top_i[kWave];
  uint64_t T;
  int n_active;
  int n_cand;
};

// Grid (G, B): block (g, b) merges row b's n lists (list p at
// part + (b*n + p)*k) and, with RESCORE, rescores the winners g*per ..
// g*per+per-1 (per = ceil(k/G), one wave each). Block g == 0 writes idx and
// score. All G blocks of a row compute the same winners.
template <typename T, bool RESCORE>
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(
    const float* __restrict__ part_s, const int* __restrict__ part_i, int n, int64_t V, int k,
    const T* __restrict__ W, const T* __restrict__ H, int d, int32_t* __restrict__ idx,
    float* __restrict__ score, float* __restrict__ logits) {
  __shared__ MergeSmem m;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t b = blockIdx.y;
  const float* ps = part_s + b * n * k;
  const int* pi = part_i + b * n * k;

  // 1. a bound T that between k and 64 heads reach (wave 0); the lists whose head reaches T
  if (wave == 0) {
    // all loads first, from clamped (valid) addresses, then the keys
    float hs[kHeadE];
    int hid[kHeadE];
#pragma unroll
    for (int e = 0; e < kHeadE; ++e) {
      const int p = min(e * kWave + lane, n - 1);
      hs[e] = ps[(int64_t)p * k];
      hid[e] = pi[(int64_t)p * k];
    }
    uint64_t key[kHeadE];
#pragma unroll
    for (int e = 0; e < kHeadE; ++e)
      key[e] = (e * kWave + lane < n && hid[e] != kSentinelId) ? cand_key(hs[e], hid[e]) : 0ull;
    const uint64_t T1 = wave_window_threshold<kHeadE>(key, k, kWave);
    int na = 0;
#pragma unroll
    for (int e = 0; e < kHeadE; ++e) {
      const bool act = key[e] != 0 && key[e] >= T1;
      const unsigned long long mk = __ballot(act);
      if (act) m.active[na + lanes_below(mk)] = e * kWave + lane;
      na += __popcll(mk);
    }
    if (lane == 0) {
      m.T = T1;
      m.n_active = na;
      m.n_cand = 0;
    }
  }
  __syncthreads();

  // 2. entries of the active lists that reach T; wave w takes active lists
  //    w, w+8, ... (at most 8 of them), all loads issued first
  {
    const uint64_t T1 = m.T;
    const int na = m.n_active;
    constexpr int kPerWave = kWave / kMergeWaves;
    const int j = min(lane, k - 1);
    float es[kPerWave];
    int ei[kPerWave];
#pragma unroll
    for (int q = 0; q < kPerWave; ++q) {
      const int a = wave + q * kMergeWaves;
      const int p = a < na ? m.active[a] : 0;
      es[q] = ps[(int64_t)p * k + j];
      ei[q] = pi[(int64_t)p * k + j];
    }
#pragma unroll
    for (int q = 0; q < kPerWave; ++q) {
      if (wave + q * kMergeWaves >= na) break;
      const uint64_t key = (lane < k && ei[q] != kSentinelId) ? cand_key(es[q], ei[q]) : 0ull;
      const bool pass = key != 0 && key >= T1;
      const unsigned long long mk = __ballot(pass);
      int base = 0;
      if (lane == 0 && mk) base = atomicAdd(&m.n_cand, __popcll(mk));
      base = __shfl(base, 0);
      const int slot = base + lanes_below(mk);
      if (pass && slot < kCandSlots) m.cand[slot] = key;
    }
  }
  __syncthreads();

  // 3. the k best candidates, in order (wave 0)
  if (wave == 0) {
    const int nc = m.n_cand;
    if (nc <= kCandSlots) {
      uint64_t key[kCandE];
#pragma unroll
      for (int e = 0; e < kCandE; ++e) {
        const int j = e * kWave + lane;
        key[e] = j < nc ? m.cand[j] : 0ull;
      }
      wave_topk_emit<kCandE>(key, k, m.tmp, m.top_s, m.top_i);
    } else {
      float s;
      int i;
      merge_lists_seq(ps, pi, n, k, s, i);
      m.top_s[lane] = s;
      m.top_i[lane] = i;
    }
    if (blockIdx.x == 0 && lane < k) {
      idx[b * k + lane] = m.top_i[lane];
      if (score) score[b * k + lane] = m.top_s[lane];
    }
  }
  if constexpr (RESCORE) {
    __syncthreads();
    const int per = (k + gridDim.x - 1) / gridDim.x;
    const int j = blockIdx.x * per + wave;
    if (wave < per && j < k) {
      const int v = m.top_i[j];
      float acc = __builtin_nanf("");
      if (v >= 0 && v < V) acc = wave_row_dot<T>(W + (int64_t)v * d, H + b * (int64_t)d, d);
      if (lane == 0) logits[b * k + j] = acc;
    }
  }
}

// ================================================================ launchers

hipError_t launch_rescore(int dtype, const void* W, const void* H, const int32_t* idx, int64_t B, int k,
                          int64_t V, int d, float* logits, hipStream_t stream) {
  const int64_t npairs = B * k;
  dim3 grid((unsigned)((npairs + 3) / 4));
  if (dtype == 0)
    hipLaunchKernelGGL(rescore_kernel<uint16_t>, grid, dim3(256), 0, stream, (const uint16_t*)W,
                       (const uint16_t*)H, idx, npairs, k, V, d, logits);
  else
    hipLaunchKernelGGL(rescore_kernel<float>, grid, dim3(256), 0, stream, (const float*)W, (const float*)H, idx,
                       npairs, k, V, d, logits);
  return hipGetLastError();
}

hipError_t launch_merge(int dtype, const float* part_s, const int* part_i, int n, int64_t V,
                        int64_t B, int k, const void* W, const void* H, int d, int32_t* idx, float* score,
                        float* logits, hipStream_t stream) {
  if (n < 1 || n > kMaxLists) return hipErrorInvalidValue;
  if (!logits) {
    dim3 grid(1, (unsigned)B);
    hipLaunchKernelGGL((merge_kernel<uint16_t, false>), grid, dim3(kMergeThreads), 0, stream, part_s, part_i, n,
                       V, k, (const uint16_t*)nullptr, (const uint16_t*)nullptr, d, idx, score, logits);
    return hipGetLastError();
  }
  dim3 grid((unsigned)((k + kMergeWaves - 1) / kMergeWaves), (unsigned)B);
  if (dtype == 0)
    hipLaunchKernelGGL((merge_kernel<uint16_t, true>), grid, dim3(kMergeThreads), 0, stream, part_s, part_i, n,
                       V, k, (const uint16_t*)W, (const uint16_t*)H, d, idx, score, logits);
  else
    hipLaunchKernelGGL((merge_kernel<float, true>), grid, dim3(kMergeThreads), 0, stream, part_s, part_i, n,
                       V, k, (const float*)W, (const float*)H, d, idx, score, logits);
  return hipGetLastError();
}

}  // namespace lrh
